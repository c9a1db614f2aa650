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

KERNEL_SOURCES = {
    "fwd_bf16": ["csrc/fa_fwd_bf16.hip", "csrc/fa_internal.h"],
    "fwd_bf16_bias": ["csrc/fa_fwd_bf16.hip", "csrc/fa_internal.h"],
    "fwd_bf16_varlen": ["csrc/fa_fwd_bf16.hip", "csrc/fa_internal.h"],
    "fwd_fp8": ["csrc/fa_fwd_fp8.hip", "csrc/fa_internal.h"],
    "fwd_f32": ["csrc/fa_fwd_f32.hip", "csrc/fa_internal.h"],
    "decode": ["csrc/fa_decode.hip", "csrc/fa_internal.h"],
    "decode_paged": ["csrc/fa_decode.hip", "csrc/fa_internal.h"],
    "bwd_pre": ["csrc/fa_bwd.hip", "csrc/fa_internal.h"],
    "bwd_dkdv": ["csrc/fa_bwd.hip", "csrc/fa_internal.h"],
    "bwd_dq": ["csrc/fa_bwd.hip", "csrc/fa_internal.h"],
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
