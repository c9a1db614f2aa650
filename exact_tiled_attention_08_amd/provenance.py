"""Identity of the kernel sources a measurement was taken with.

A stored counter measurement is valid only for the kernel code it was taken on; the hash
below changes whenever that code changes (comments and layout do not count), and
consumers then treat the stored figure as absent.
"""
from __future__ import annotations

import hashlib
import os
import re

PKG = os.path.dirname(os.path.abspath(__file__))

# Each kind's kernel source, the shared device header, and the host file that sets its
# launch (grid, block -> tile mapping): a change to any of them can change what the counters
# read.
_COMMON = ["csrc/fa_internal.h", "csrc/fa_api.hip"]
KERNEL_SOURCES = {
    "fwd_bf16": ["csrc/fa_fwd_bf16.hip", *_COMMON],
    "fwd_bf16_bias": ["csrc/fa_fwd_bf16.hip", *_COMMON],
    "fwd_bf16_varlen": ["csrc/fa_fwd_bf16.hip", *_COMMON],
    "fwd_fp8": ["csrc/fa_fwd_fp8.hip", *_COMMON],
    "fwd_f32": ["csrc/fa_fwd_f32.hip", *_COMMON],
    "decode": ["csrc/fa_decode.hip", *_COMMON],
    "decode_paged": ["csrc/fa_decode.hip", *_COMMON],
    "bwd_pre": ["csrc/fa_bwd.hip", *_COMMON],
    "bwd_dkdv": ["csrc/fa_bwd.hip", *_COMMON],
    "bwd_dq": ["csrc/fa_bwd.hip", *_COMMON],
}


_COMMENT = re.compile(r"/\*.*?\*/|//[^\n]*", re.S)


def code_text(text: str) -> str:
    """The code of a C/C++/HIP source with its comments removed and every run of white space
    reduced to one blank: edits to comments or layout leave it unchanged. (The kernel
    sources hold no string literal with a comment marker in it.)"""
    return " ".join(_COMMENT.sub(" ", text).split())


def source_hash(kind: str) -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES[kind]:
        with open(os.path.join(PKG, rel), encoding="utf-8") as f:
            h.update(code_text(f.read()).encode())
        h.update(b"\0")
    return h.hexdigest()[:16]
