"""Digest of the sources libhxq.so is built from.

The build embeds it in the library (hxq_source_digest()); the binding
recomputes it from the files in the tree and refuses a library built from
other sources, so a stale build is never timed or tested by mistake."""

from __future__ import annotations

import hashlib
import os

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
HEADER = os.path.join(os.path.dirname(HERE), "include", "hxq.h")


def source_files():
    names = sorted(f for f in os.listdir(CSRC) if f.endswith((".hip", ".cpp", ".h")))
    return [os.path.join(CSRC, f) for f in names] + [HEADER]


def source_digest() -> str:
    """SHA-256 over the names and bytes of the kernel and host sources and the
    public header, first 32 hex digits."""
    h = hashlib.sha256()
    for path in source_files():
        h.update(os.path.basename(path).encode() + b"\0")
        with open(path, "rb") as f:
            h.update(f.read())
        h.update(b"\0")
    return h.hexdigest()[:32]
