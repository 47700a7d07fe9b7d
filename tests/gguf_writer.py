"""A minimal GGUF writer for tests, written from the layout the pages give
("GGUF Inferencer in R", section 2.1 byte blueprint; "GGUF: The File Format
Powering Local LLM Inference", what is stored inside a GGUF file): header,
metadata entries, tensor records, zero padding to the alignment, data. It is
independent of the library's reader, which the tests check against it."""

from __future__ import annotations

import struct

SCALAR = {0: "<B", 1: "<b", 2: "<H", 3: "<h", 4: "<I", 5: "<i", 6: "<f", 7: "<?",
          10: "<Q", 11: "<q", 12: "<d"}
STRING, ARRAY = 8, 9


def gstr(text) -> bytes:
    b = text.encode() if isinstance(text, str) else bytes(text)
    return struct.pack("<Q", len(b)) + b


def value(vtype: int, v) -> bytes:
    if vtype in SCALAR:
        return struct.pack(SCALAR[vtype], v)
    if vtype == STRING:
        return gstr(v)
    if vtype == ARRAY:
        etype, items = v
        out = struct.pack("<IQ", etype, len(items))
        for it in items:
            out += value(etype, it)
        return out
    raise ValueError(vtype)


def gguf_bytes(kvs, tensors, alignment=32, version=3):
    """kvs: [(key, vtype, value)]; tensors: [(name, dims fastest first, type, data bytes)].
    Tensor data is laid out back to back, each at a multiple of `alignment`.
    Returns (file bytes, data start, [relative offsets])."""
    out = b"GGUF" + struct.pack("<IQQ", version, len(tensors), len(kvs))
    for key, vtype, v in kvs:
        out += gstr(key) + struct.pack("<I", vtype) + value(vtype, v)
    offs, rel = [], 0
    for name, dims, ttype, data in tensors:
        offs.append(rel)
        out += gstr(name) + struct.pack("<I", len(dims))
        out += b"".join(struct.pack("<Q", d) for d in dims)
        out += struct.pack("<IQ", ttype, rel)
        rel += len(data)
        rel += -rel % alignment
    out += b"\0" * (-len(out) % alignment)
    start = len(out)
    for (name, dims, ttype, data), off in zip(tensors, offs):
        out += b"\0" * (start + off - len(out))
        out += bytes(data)
    return out, start, offs
