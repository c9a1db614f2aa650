"""Float64 CPU oracle for exact attention (TEST INFRASTRUCTURE ONLY).

Only the test suite, the smoke check in ``__graft_entry__`` and the CPU-baseline
leg of ``bench.py`` may import this package. The HIP library never imports,
links or calls it, and it imports nothing from the HIP library: the two share
only the seeded input generators in ``workloads.py``.

``attention`` evaluates the plain definition O = softmax(Q K^T * scale + mask) V
row by row in double precision (the C source states each passage it follows), with an
optional additive bias on the scaled scores;
``attention_bwd`` evaluates the gradients of sum(O * dO) with respect to Q, K, V (and,
with a bias, with respect to a full bias) from the same definition by the chain rule. ``paged_attention`` is the same definition
for one query per sequence whose keys and values live in a paged cache: it first
gathers each sequence's logical key/value rows through its block table, then calls
``attention``. ``attention_varlen`` applies the definition to each sequence of a packed
batch of variable-length sequences.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

F32 = 1
BF16 = 0
F64 = 2

_lib = None


def build(force: bool = True) -> str:
    """Compile oracle.c into liboracle.so with gcc (plain C, OpenMP)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.check_call(
            ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def load_library(path: str):
    """Open a compiled oracle library and declare its entry point."""
    lib = ctypes.CDLL(path)
    f = lib.oracle_attention
    f.restype = ctypes.c_int
    f.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int,
                  ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                  ctypes.c_double, ctypes.c_int,
                  ctypes.c_void_p, ctypes.c_longlong, ctypes.c_int,
                  ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    fb = lib.oracle_attention_bias
    fb.restype = ctypes.c_int
    fb.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int,
                   ctypes.c_void_p, ctypes.c_int, ctypes.c_longlong, ctypes.c_longlong,
                   ctypes.c_longlong,
                   ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                   ctypes.c_double, ctypes.c_int,
                   ctypes.c_void_p, ctypes.c_longlong, ctypes.c_int,
                   ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    g = lib.oracle_attention_bwd
    g.restype = ctypes.c_int
    g.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int,
                  ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                  ctypes.c_double, ctypes.c_int,
                  ctypes.c_void_p, ctypes.c_longlong, ctypes.c_void_p, ctypes.c_longlong,
                  ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    gb = lib.oracle_attention_bwd_bias
    gb.restype = ctypes.c_int
    gb.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int,
                   ctypes.c_void_p, ctypes.c_int, ctypes.c_longlong, ctypes.c_longlong,
                   ctypes.c_longlong,
                   ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                   ctypes.c_double, ctypes.c_int,
                   ctypes.c_void_p, ctypes.c_longlong, ctypes.c_void_p, ctypes.c_longlong,
                   ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                   ctypes.c_void_p]
    return lib


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=False)
        _lib = load_library(_LIB)
    return _lib


def default_threads() -> int:
    """Host cores this process may use, capped at 16 (the CPU share of one GPU)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _as_input(x):
    """Return (contiguous ndarray holding the raw element bits, dtype code)."""
    try:
        import torch
        if isinstance(x, torch.Tensor):
            x = x.detach().cpu().contiguous()
            if x.dtype == torch.bfloat16:
                return x.view(torch.int16).numpy().view(np.uint16), BF16
            if x.dtype == torch.float32:
                return x.numpy(), F32
            if x.dtype == torch.float64:
                return x.numpy(), F64
            raise TypeError(f"oracle inputs must be float32, bfloat16 or float64, got {x.dtype}")
    except ImportError:  # pragma: no cover
        pass
    x = np.ascontiguousarray(x)
    if x.dtype == np.float32:
        return x, F32
    if x.dtype == np.float64:
        return x, F64
    if x.dtype == np.uint16:  # raw bfloat16 bits
        return x, BF16
    raise TypeError(f"oracle inputs must be float32 or raw bfloat16 (uint16), got {x.dtype}")


def _causal_code(causal) -> int:
    """0 = no mask, 1 (or True) = causal with the queries at the end of the key sequence
    (bottom-right), 2 = causal with the queries at its start (top-left)."""
    c = int(causal)
    if c not in (0, 1, 2):
        raise ValueError("causal must be 0/False, 1/True (bottom-right) or 2 (top-left)")
    return c


def _bias_view(bias, B: int, H: int, Nq: int, Nk: int):
    """(tensor kept alive, dtype code, (sb, sh, sq)) for a CPU bias tensor broadcastable
    to [B, H, Nq, Nk]: element (b, h, i, j) is at b*sb + h*sh + i*sq + j of the tensor's
    data (a broadcast dimension gets stride 0)."""
    import torch
    bt = torch.as_tensor(bias).detach().cpu()
    if bt.dtype not in (torch.bfloat16, torch.float32, torch.float64):
        raise TypeError(f"bias must be bfloat16, float32 or float64, got {bt.dtype}")
    while bt.dim() < 4:
        bt = bt.unsqueeze(0)
    if bt.dim() != 4:
        raise ValueError("bias must broadcast to [B, H, Nq, Nk]")
    if bt.shape[3] != Nk or bt.stride(3) != 1:   # keys must be contiguous: spell them out
        bt = bt.expand(*bt.shape[:3], Nk).contiguous()
    be = bt.expand(B, H, Nq, Nk)                  # raises if not broadcastable
    code = {torch.bfloat16: BF16, torch.float32: F32, torch.float64: F64}[bt.dtype]
    return be, code, tuple(int(x) for x in be.stride()[:3])


def attention(q, k, v, scale: float, causal: bool = False, rows=None,
              want_p: bool = False, threads: int | None = None, bias=None):
    """Float64 attention for q [B,H,Nq,d], k/v [B,H,Nk,d] (float32, bfloat16 or float64;
    float64 carries exactly dequantized 8-bit inputs).

    ``causal``: 0/False none; 1/True the query rows are the last Nq key positions (query i
    sees key j iff j <= i + Nk - Nq); 2 they are the first Nq (j <= i).

    ``rows``: optional flat row ids (b*H + h)*Nq + i to evaluate (sampled
    checks); default all rows. ``scale`` is used as the exact double given;
    callers pass the float32-rounded value the kernel receives.
    ``bias``: optional CPU tensor (bfloat16, float32 or float64) broadcastable to
    [B, H, Nq, Nk], added to the scaled scores of visible pairs (-inf hides a key).
    Returns (o [nrows, d] float64, lse [nrows] float64[, p [nrows, Nk]]).
    """
    qa, dt = _as_input(q)
    ka, dtk = _as_input(k)
    va, dtv = _as_input(v)
    if not (dt == dtk == dtv):
        raise TypeError("q, k and v must share one dtype")
    if qa.ndim != 4 or ka.ndim != 4 or va.ndim != 4:
        raise ValueError("q, k, v must be [B, H, N, d]")
    B, H, Nq, d = qa.shape
    if ka.shape[:2] != (B, H) or ka.shape[3] != d or va.shape != ka.shape:
        raise ValueError("k and v must be [B, H, Nk, d] matching q")
    Nk = ka.shape[2]
    if rows is None:
        rows_arr = None
        nrows = B * H * Nq
    else:
        rows_arr = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
        nrows = int(rows_arr.size)
    threads = threads or default_threads()
    o = np.empty((nrows, d), np.float64)
    lse = np.empty((nrows,), np.float64)
    p = np.empty((nrows, Nk), np.float64) if want_p else None
    scratch = np.empty((threads, Nk), np.float64)
    tail = (float(scale), _causal_code(causal),
            rows_arr.ctypes.data if rows_arr is not None else None, nrows, threads,
            scratch.ctypes.data, o.ctypes.data, lse.ctypes.data,
            p.ctypes.data if p is not None else None)
    if bias is None:
        rc = _load().oracle_attention(qa.ctypes.data, ka.ctypes.data, va.ctypes.data, dt,
                                      B, H, Nq, Nk, d, *tail)
    else:
        bt, bcode, (sb, sh, sq) = _bias_view(bias, B, H, Nq, Nk)
        rc = _load().oracle_attention_bias(qa.ctypes.data, ka.ctypes.data, va.ctypes.data, dt,
                                           bt.data_ptr(), bcode, sb, sh, sq,
                                           B, H, Nq, Nk, d, *tail)
    if rc != 0:
        raise ValueError("oracle_attention rejected its arguments")
    return (o, lse, p) if want_p else (o, lse)


def attention_bwd(q, k, v, do, scale: float, causal: bool = False, qrows=None, krows=None,
                  threads: int | None = None, bias=None, want_dbias: bool = False):
    """Float64 gradients of sum(O * dO) for O = attention(q, k, v[, bias]).

    q, do [B,H,Nq,d]; k, v [B,H,Nk,d]; all float32, all bfloat16 or all float64.
    ``qrows``: flat query rows (b*H + h)*Nq + i whose dQ is returned (default all);
    ``krows``: flat key rows (b*H + h)*Nk + j whose dK and dV are returned (default all).
    ``bias``: optional CPU tensor broadcastable to [B, H, Nq, Nk], added to the scaled
    scores as in ``attention``; with ``want_dbias`` the gradient with respect to a full
    [B, H, Nq, Nk] bias is returned too (dL/dbias = dS; every query row, qrows None).
    Returns (dq [nq, d], dk [nk, d], dv [nk, d]) float64, and dbias [B*H*Nq, Nk] float64
    when want_dbias.
    """
    qa, dt = _as_input(q)
    ka, dtk = _as_input(k)
    va, dtv = _as_input(v)
    da, dtd = _as_input(do)
    if not (dt == dtk == dtv == dtd):
        raise TypeError("q, k, v and do must share one dtype")
    if qa.ndim != 4 or ka.ndim != 4 or va.ndim != 4 or da.shape != qa.shape:
        raise ValueError("q, do must be [B, H, Nq, d] and k, v [B, H, Nk, d]")
    B, H, Nq, d = qa.shape
    if ka.shape[:2] != (B, H) or ka.shape[3] != d or va.shape != ka.shape:
        raise ValueError("k and v must be [B, H, Nk, d] matching q")
    Nk = ka.shape[2]

    def rows_of(rows, total):
        if rows is None:
            return None, total
        arr = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
        return arr, int(arr.size)

    qr, nq = rows_of(qrows, B * H * Nq)
    kr, nk = rows_of(krows, B * H * Nk)
    threads = threads or default_threads()
    dq = np.empty((nq, d), np.float64)
    dk = np.empty((nk, d), np.float64)
    dv = np.empty((nk, d), np.float64)
    rows_args = (qr.ctypes.data if qr is not None else None, nq,
                 kr.ctypes.data if kr is not None else None, nk, threads,
                 dq.ctypes.data, dk.ctypes.data, dv.ctypes.data)
    if bias is None:
        if want_dbias:
            raise ValueError("want_dbias needs a bias")
        rc = _load().oracle_attention_bwd(
            qa.ctypes.data, ka.ctypes.data, va.ctypes.data, da.ctypes.data, dt, B, H, Nq, Nk, d,
            float(scale), _causal_code(causal), *rows_args)
        if rc != 0:
            raise ValueError("oracle_attention_bwd rejected its arguments")
        return dq, dk, dv
    bt, bcode, (sb, sh, sq) = _bias_view(bias, B, H, Nq, Nk)
    db = np.empty((B * H * Nq, Nk), np.float64) if want_dbias else None
    rc = _load().oracle_attention_bwd_bias(
        qa.ctypes.data, ka.ctypes.data, va.ctypes.data, da.ctypes.data, dt, bt.data_ptr(), bcode,
        sb, sh, sq, B, H, Nq, Nk, d, float(scale), _causal_code(causal), *rows_args,
        db.ctypes.data if db is not None else None)
    if rc != 0:
        raise ValueError("oracle_attention_bwd_bias rejected its arguments")
    return (dq, dk, dv, db) if want_dbias else (dq, dk, dv)


def paged_gather(cache, block_table, seq_len: int, b: int, page_size: int):
    """Logical rows of sequence b from a paged cache, as [H, seq_len, d].

    cache [num_pages, page_size, H, d]; block_table [B, max_pages] (int). The key at
    logical position t of sequence b is cache[block_table[b, t // page_size], t % page_size]
    (the page indirection of a paged key/value cache; "FlashAttention: Attention Is Limited
    by Memory, Not Math", section "Where it helps, and where it does not", names engines
    that pair split-KV decoding with paged caches). A page id outside [0, num_pages) holds
    no keys: its positions are left out.
    """
    import torch
    num_pages = cache.shape[0]
    pieces = []
    for j in range(-(-seq_len // page_size)):            # logical page j: positions j*ps ..
        n = min(page_size, seq_len - j * page_size)
        page = int(block_table[b, j])
        if 0 <= page < num_pages:
            pieces.append(cache[page, :n])                # [n, H, d]
    if not pieces:
        return cache.new_zeros((cache.shape[2], 0, cache.shape[3]))
    return torch.cat(pieces, dim=0).permute(1, 0, 2).contiguous()   # [H, n, d]


def paged_attention(q, k_cache, v_cache, block_table, seq_lens, page_size: int, scale: float,
                    threads: int | None = None):
    """Float64 attention of one query per (b, h) over a paged cache.

    q [B, H, 1, d]; k_cache, v_cache [num_pages, page_size, H, d] (float32 or bfloat16,
    CPU tensors); block_table [B, max_pages] and seq_lens [B] (integers). Sequence b
    attends to its first seq_lens[b] logical positions (all visible: one query at the end
    of its sequence). Returns (o [B*H, d], lse [B*H]) float64; a sequence with no key
    gets O = 0 and LSE = -inf.
    """
    B, H, nq, d = q.shape
    if nq != 1:
        raise ValueError("paged_attention takes one query per (b, h)")
    o = np.zeros((B * H, d), np.float64)
    lse = np.full((B * H,), -np.inf, np.float64)
    for b in range(B):
        kb = paged_gather(k_cache, block_table, int(seq_lens[b]), b, page_size)
        vb = paged_gather(v_cache, block_table, int(seq_lens[b]), b, page_size)
        if kb.shape[1] == 0:
            continue
        ob, lb = attention(q[b:b + 1], kb[None], vb[None], scale, False, threads=threads)
        o[b * H:(b + 1) * H] = ob
        lse[b * H:(b + 1) * H] = lb
    return o, lse


def attention_varlen(q, k, v, cu_seqlens_q, cu_seqlens_k, scale: float, causal: bool = False,
                     threads: int | None = None):
    """Float64 attention of a packed batch of variable-length sequences.

    q [total_q, H, d]; k, v [total_k, H, d] (float32 or bfloat16, CPU); cu_seqlens_q and
    cu_seqlens_k: B + 1 non-decreasing integers from 0. Sequence b's query rows
    cu_seqlens_q[b] .. cu_seqlens_q[b+1]-1 attend to its key rows cu_seqlens_k[b] ..
    cu_seqlens_k[b+1]-1 of the same head, and to nothing else, with the mask of
    ``attention`` taken inside the sequence (causal: query i of a sequence of nq queries
    and nk keys sees key j iff j <= i + nk - nq; "Explain FlashAttention ...", section
    "Executable recurrence, with an empty-state policy": positions are absolute within
    the sequence). Returns (o [total_q, H, d], lse [H, total_q]) float64; a query row with
    no visible key gets O = 0 and LSE = -inf.
    """
    total_q, H, d = q.shape
    cq = [int(x) for x in cu_seqlens_q]
    ck = [int(x) for x in cu_seqlens_k]
    if len(cq) != len(ck) or cq[0] != 0 or ck[0] != 0 or cq[-1] != total_q or ck[-1] != k.shape[0]:
        raise ValueError("cu_seqlens must start at 0 and end at the packed lengths")
    o = np.zeros((total_q, H, d), np.float64)
    lse = np.full((H, total_q), -np.inf, np.float64)
    for b in range(len(cq) - 1):
        nq, nk = cq[b + 1] - cq[b], ck[b + 1] - ck[b]
        if nq < 0 or nk < 0:
            raise ValueError("cu_seqlens must be non-decreasing")
        if nq == 0 or nk == 0:
            continue  # no rows, or rows that see no key (O = 0, LSE = -inf)
        qb = q[cq[b]:cq[b + 1]].permute(1, 0, 2)[None].contiguous()   # [1, H, nq, d]
        kb = k[ck[b]:ck[b + 1]].permute(1, 0, 2)[None].contiguous()
        vb = v[ck[b]:ck[b + 1]].permute(1, 0, 2)[None].contiguous()
        ob, lb = attention(qb, kb, vb, scale, causal, threads=threads)
        o[cq[b]:cq[b + 1]] = ob.reshape(H, nq, d).transpose(1, 0, 2)
        lse[:, cq[b]:cq[b + 1]] = lb.reshape(H, nq)
    return o, lse


def attention_varlen_bwd(q, k, v, do, cu_seqlens_q, cu_seqlens_k, scale: float,
                         causal: bool = False, threads: int | None = None):
    """Float64 gradients of sum(O * dO) for O = attention_varlen(q, k, v, ...).

    q, do [total_q, H, d]; k, v [total_k, H, d] (float32 or bfloat16, CPU), with the
    sequence offsets and the in-sequence mask of ``attention_varlen``. The sequences share no
    scores, so the gradients are those of ``attention_bwd`` on each sequence's slice (the
    chain rule of "Explain FlashAttention ...", section "Exact attention, finite precision
    and backward", applied per sequence). Returns (dq [total_q, H, d], dk [total_k, H, d],
    dv [total_k, H, d]) float64; rows of a sequence with no query rows or no keys are zero.
    """
    total_q, H, d = q.shape
    cq = [int(x) for x in cu_seqlens_q]
    ck = [int(x) for x in cu_seqlens_k]
    if len(cq) != len(ck) or cq[0] != 0 or ck[0] != 0 or cq[-1] != total_q or ck[-1] != k.shape[0]:
        raise ValueError("cu_seqlens must start at 0 and end at the packed lengths")
    if do.shape != q.shape or v.shape != k.shape:
        raise ValueError("do must match q and v must match k")
    dq = np.zeros((total_q, H, d), np.float64)
    dk = np.zeros((k.shape[0], H, d), np.float64)
    dv = np.zeros((k.shape[0], H, d), np.float64)
    for b in range(len(cq) - 1):
        nq, nk = cq[b + 1] - cq[b], ck[b + 1] - ck[b]
        if nq < 0 or nk < 0:
            raise ValueError("cu_seqlens must be non-decreasing")
        if nq == 0 or nk == 0:
            continue  # nothing attends: every gradient of the sequence is zero
        sl = lambda t, lo, hi: t[lo:hi].permute(1, 0, 2)[None].contiguous()   # [1, H, n, d]
        gq, gk, gv = attention_bwd(sl(q, cq[b], cq[b + 1]), sl(k, ck[b], ck[b + 1]),
                                   sl(v, ck[b], ck[b + 1]), sl(do, cq[b], cq[b + 1]),
                                   scale, causal, threads=threads)
        dq[cq[b]:cq[b + 1]] = gq.reshape(H, nq, d).transpose(1, 0, 2)
        dk[ck[b]:ck[b + 1]] = gk.reshape(H, nk, d).transpose(1, 0, 2)
        dv[ck[b]:ck[b + 1]] = gv.reshape(H, nk, d).transpose(1, 0, 2)
    return dq, dk, dv
