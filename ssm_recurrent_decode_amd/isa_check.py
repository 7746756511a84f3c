"""Scan the device assembly of this library for instruction classes it must never
contain: stores and atomics through the scalar data cache, and that cache's
write-back/discard.  Every write here goes through vector memory instructions.
Run by build.py after compiling; raises on a hit."""
from __future__ import annotations

import re

_FORBIDDEN = re.compile(
    r"^\s*(s_store_|s_buffer_store|s_scratch_store|s_atomic_|s_buffer_atomic|"
    r"s_dcache_wb|s_dcache_discard)", re.MULTILINE)


def check(asm_files) -> None:
    hits = []
    for path in asm_files:
        with open(path) as f:
            text = f.read()
        for m in _FORBIDDEN.finditer(text):
            line = text[m.start(): text.find("\n", m.start())]
            hits.append(f"{path}: {line.strip()}")
    if hits:
        raise RuntimeError("forbidden scalar-cache write instructions in device code:\n" +
                           "\n".join(hits[:20]))
